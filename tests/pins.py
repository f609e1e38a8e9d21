"""Independent checks that pin the oracle (shared by the oracle tests and the
mutation tests, which plant mistakes in the oracle and expect these to fail).

Nothing here reuses the oracle's arithmetic:
* E4M3 and E8M0 values come from torch's own dtype casts (library routines);
* E2M1 values come from the hand-typed OCP table in ``golden/e2m1_grid.txt``;
* scores are exact rationals (``fractions.Fraction``) from pure-Python loops
  over the page bytes, written from the page layout reading;
* the selection is a Python sort / a heap.
"""

import heapq
import json
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_e2m1():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_grid.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    return vals


def golden_e4m3_points():
    pts = {}
    with open(os.path.join(GOLDEN, "e4m3fn_points.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            pts[int(c, 16)] = float(v)
    return pts


def golden_mxfp4_blocks():
    cases = []
    with open(os.path.join(GOLDEN, "mxfp4_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b, c = line.split(";")
            cases.append((np.array([float(x) for x in a.split()]), int(b),
                          np.array([int(x) for x in c.split()])))
    return cases


def hand_example():
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        return json.load(f)


def torch_e4m3(codes):
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(codes, dtype=np.uint8)))
    return t.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def torch_e8m0(codes):
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(codes, dtype=np.uint8)))
    return t.view(torch.float8_e8m0fnu).float().numpy().astype(np.float64)


class Exact:
    """Exact-rational reader of the page bytes (the layout reading restated as
    loops: token t at byte 68t; dim d in byte d//2, low nibble for even d;
    scale of dim d at byte 64 + d//32)."""

    def __init__(self):
        g = golden_e2m1()
        self.e2m1 = [Fraction(g[c]) for c in range(16)]
        self.e4m3 = [Fraction(float(v)) if np.isfinite(v) else None
                     for v in torch_e4m3(np.arange(256))]
        self.e8m0 = [Fraction(float(v)) if np.isfinite(v) else None
                     for v in torch_e8m0(np.arange(256))]

    def token(self, page, t):
        base = 68 * t
        out = []
        for d in range(128):
            byte = int(page[base + d // 2])
            nib = (byte & 0xF) if d % 2 == 0 else (byte >> 4)
            out.append(self.e2m1[nib] * self.e8m0[int(page[base + 64 + d // 32])])
        return out

    def page_score(self, page, q, ntok=128):
        """max over tokens t < ntok of q . k_t, exactly."""
        best = None
        for t in range(ntok):
            k = self.token(page, t)
            s = sum((qa * kb for qa, kb in zip(q, k)), Fraction(0))
            best = s if best is None or s > best else best
        return best

    def run(self, q_codes, pool, block_table, req_of_row, pos_of_row, scale, q_dtype="e4m3"):
        """Exact 16-slot output of every row: returns (out [T,H,16], scores).
        Index-Q values come from torch's own casts (E4M3 bytes or bfloat16
        bit patterns)."""
        q_codes = np.asarray(q_codes)
        if q_dtype == "bf16":
            qv = torch.from_numpy(np.ascontiguousarray(q_codes.astype(np.uint16)).view(np.int16))
            qv = qv.view(torch.bfloat16).double().numpy()
            q_of = lambda row, h: [Fraction(float(v)) for v in qv[row, h]]
        else:
            q_of = lambda row, h: [self.e4m3[int(c)] for c in q_codes[row, h]]
        T, H, _ = q_codes.shape
        pool = np.asarray(pool, dtype=np.uint8).reshape(-1, 8704)
        out = np.full((T, H, 16), -1, dtype=np.int64)
        scores = {}
        cache = {}
        for row in range(T):
            p = int(pos_of_row[row])
            if p < 0:
                continue
            L = p // 128
            r = int(req_of_row[row])
            for h in range(H):
                q = q_of(row, h)
                key = tuple(int(c) for c in q_codes[row, h])
                s = []
                for j in range(L):
                    phys = int(block_table[r][j])
                    ck = (key, phys)
                    if ck not in cache:
                        cache[ck] = self.page_score(pool[phys], q)
                    s.append(Fraction(scale) * cache[ck])
                ranked = sorted(range(L), key=lambda j: (-s[j], j))
                n = min(15, L)
                out[row, h, :n] = ranked[:n]
                out[row, h, 15] = L
                scores[(row, h)] = s
        return out, scores


def heap_select(scores, L):
    """Top-15 by a heap: largest score, then smallest id."""
    best = heapq.nlargest(min(15, L), range(L), key=lambda j: (scores[j], -j))
    out = [-1] * 16
    out[:len(best)] = best
    out[15] = L
    return out


def check_invariants(out, L):
    """The contract every (row, head) output must satisfy, given its L."""
    out = np.asarray(out)
    T, H, _ = out.shape
    for t in range(T):
        for h in range(H):
            o = out[t, h]
            if L[t] < 0:
                assert np.all(o == -1), (t, h, o)
                continue
            assert o[15] == L[t], (t, h, o, L[t])
            n = min(15, int(L[t]))
            ids = o[:n]
            assert np.all(o[n:15] == -1), (t, h, o)
            assert np.all((ids >= 0) & (ids < L[t])), (t, h, o)
            assert len(set(ids.tolist())) == n, (t, h, o)
            if L[t] <= 15:
                assert set(ids.tolist()) == set(range(int(L[t]))), (t, h, o)
