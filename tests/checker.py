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
  GPU's pick is also a valid tie.
Returns the fraction of (row, head) outputs that match bit-exactly.
"""

import numpy as np

REL_TOL = 1e-4


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
                tol = rel_tol * (np.abs(s).max() if s.size else 0.0)
                sg = s[ids]
                so = s[o[:n]]
                bad = np.abs(sg - so) > tol
                assert not bad.any(), (
                    f"row {t} head {h}: gpu {g[:n]} vs oracle {o[:n]}; score gaps "
                    f"{(sg - so)[bad]} exceed tol {tol}")
            if gpu_scores is not None and Lt > 0:
                s = np.asarray(scores[t][h], dtype=np.float64)
                tol = rel_tol * np.abs(s).max()
                gs = np.asarray(gpu_scores[t, h, :Lt], dtype=np.float64)
                diff = np.abs(gs - s)
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
            tol = rel_tol * (np.abs(s).max() if s.size else 0.0)
            sg = np.sort(s[gm])[::-1]
            so = np.sort(s[om])[::-1]
            bad = np.abs(sg - so) > tol
            assert not bad.any(), (f"row {t} head {h}: gpu {g} vs oracle {o}; score gaps "
                                   f"{(sg - so)[bad]} exceed tol {tol}")
    return exact / max(total, 1)
