"""Seeded synthetic workloads of the lightning indexer.

Shared by the oracle side (tests) and the GPU side (tests, bench).  This module
holds no arithmetic of the method: it draws random numbers, lays out requests,
pages and the block table, and casts index-Q to E4M3 with torch's own cast (a
library routine).  It never quantises K: each side writes the MXFP4 pages with
its own encoder from the fp32 K rows drawn here.

Recipe (every draw from ``numpy.random.default_rng`` with a seed list):
* sequence lengths: uniform integers in the workload's range
  (``[seed, 0]`` stream);
* every request owns ``ceil(seq_len / 128)`` logical pages; the pool holds them
  plus ``SPARE_PAGES`` spare pages, all placed by one random permutation of
  the physical ids (``[seed, 3]``), so logical and physical order differ;
* block-table entries past a request's pages point at a spare page; the whole
  pool starts filled with a poison pattern (tokens of code +6 / -6 under the
  E8M0 scale 2^113), so any read outside a row's causal history would score
  near 2^116 and surface in the selection;
* K rows of request ``r``: N(0,1) fp32, ``[seed, 1, r]`` stream, one row per
  token position below ``seq_len``;
* index-Q: N(0,1) fp32 ``[T, H, 128]`` (``[seed, 2]``), cast to
  ``torch.float8_e4m3fn``;
* planted pages (the multi-token decode workload): in each decode request a
  seeded 5 % of its history pages (at least one) get one seeded token moved by
  three standard deviations of K (sigma = 1) on every coordinate, each
  coordinate in the direction of the sign of the sum of the unit vectors of
  the request's (decoded) query rows; that lifts the token's q.k well above
  every unplanted page maximum for each row of the request, so the top-k has
  clear winners (``[seed, 4, r]``).
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

PAGE_TOKENS = 128
HEAD_DIM = 128
TOKEN_BYTES = 68
PAGE_BYTES = PAGE_TOKENS * TOKEN_BYTES
SPARE_PAGES = 3

# Poison token record: 64 code bytes then 4 scale bytes.
_POISON_POS = np.array([0x77] * 64 + [0xF0] * 4, dtype=np.uint8)   # +6 everywhere
_POISON_NEG = np.array([0xFF] * 64 + [0xF0] * 4, dtype=np.uint8)   # -6 everywhere


def poison_page():
    """One page of poison records: tokens 0..63 positive, 64..127 negative."""
    p = np.empty((PAGE_TOKENS, TOKEN_BYTES), dtype=np.uint8)
    p[:64] = _POISON_POS
    p[64:] = _POISON_NEG
    return p.reshape(PAGE_BYTES)


# name -> parameters.  The five full-size workloads, then small variants that
# the oracle finishes in seconds (parity cases) and edge cases.
CONFIGS = {
    # full sizes
    "tiny_decode": dict(decode=dict(seq_lens=[1000, 2100], query_len=1), H=1),
    "decode_batch": dict(decode=dict(R=64, lo=8192, hi=32768, query_len=1), H=1),
    "multi_token_decode": dict(decode=dict(R=128, lo=65536, hi=131072, query_len=4),
                               H=1, planted=0.05),
    "ragged_prefill": dict(prefill=dict(R=8, new=4096, ctx_lo=0, ctx_hi=61440), H=4,
                           budget=1024),
    "mixed_step": dict(decode=dict(R=32, lo=196608, hi=262144, query_len=2),
                       prefill=dict(R=2, new=8192, ctx_lo=131072, ctx_hi=131072), H=4),
    # small parity variants (same structure, oracle-sized)
    "decode_batch_small": dict(decode=dict(R=12, lo=300, hi=6000, query_len=1), H=1),
    "multi_token_small": dict(decode=dict(R=10, lo=900, hi=9000, query_len=4), H=1,
                              planted=0.05),
    "ragged_prefill_small": dict(prefill=dict(R=3, new=300, ctx_lo=0, ctx_hi=3000), H=4,
                                 budget=20),
    "mixed_small": dict(decode=dict(R=6, lo=2000, hi=9000, query_len=2),
                        prefill=dict(R=2, new=333, ctx_lo=1500, ctx_hi=4000), H=4),
    # edge cases
    "edge_short": dict(decode=dict(seq_lens=[0, 1, 2, 127, 128, 129, 255, 256, 257,
                                             1921, 2049, 2050], query_len=3), H=2),
    "edge_wide": dict(decode=dict(seq_lens=[5000, 3, 17000, 2100], query_len=8), H=8),
    "edge_prefill": dict(prefill=dict(ctx=[0, 0, 127, 1, 1919, 5000],
                                      new=[1, 130, 2, 300, 257, 64]), H=3, budget=8),
    "edge_heads5": dict(decode=dict(R=5, lo=1, hi=7000, query_len=5), H=5),
    # prefill requests with no new rows between others (empty query ranges)
    "edge_prefill_empty": dict(prefill=dict(ctx=[300, 0, 5000, 77, 2048],
                                            new=[0, 5, 0, 129, 0]), H=4, budget=0),
    # prefill tiles of 256 rows (one head) and 32 rows (eight heads)
    "prefill_h1_small": dict(prefill=dict(R=2, new=300, ctx_lo=0, ctx_hi=3000), H=1, budget=0),
    "prefill_h8_small": dict(prefill=dict(R=3, new=100, ctx_lo=500, ctx_hi=4000), H=8, budget=0),
    # more row tiles (300) than the device has workgroups: work lists of
    # several pieces, whole tiles and page ranges of split tiles mixed
    "prefill_many_tiles": dict(prefill=dict(R=6, new=3200, ctx_lo=0, ctx_hi=2000), H=4,
                               budget=0),
    # one long tile among 300 short ones (more tiles than lists): the long
    # tile is split into page ranges that join lists already holding short
    # tiles (merges inside multi-piece lists)
    "prefill_split_small": dict(prefill=dict(ctx=[0, 0, 0, 0, 0, 30000],
                                             new=[3840, 3840, 3840, 3840, 3840, 64]), H=4,
                                budget=0),
    # monotone-score cases (tests give them constructed K and Q; see
    # tests/test_gpu_trends.py): long histories in which every page is, or
    # no page after the first 15 is, a new top-15 entry
    "trend_decode": dict(decode=dict(R=5, lo=20000, hi=30000, query_len=3), H=2),
    "trend_prefill": dict(prefill=dict(R=2, new=200, ctx_lo=25000, ctx_hi=30000), H=4),
}


@dataclass
class Workload:
    name: str
    seed: int
    H: int
    query_len: int                    # decode queries per request (0: none)
    dec_seq_lens: np.ndarray          # [Rd] int32
    pre_ctx: np.ndarray               # [Rp] int32, tokens before the chunk
    pre_new: np.ndarray               # [Rp] int32, query rows of the chunk
    planted: float = 0.0
    budget: Optional[int] = None
    # derived
    seq_lens: np.ndarray = field(default=None)      # [R] decode then prefill
    n_pages: np.ndarray = field(default=None)       # [R] logical pages owned
    page_off: np.ndarray = field(default=None)      # [R] first logical slot
    phys: np.ndarray = field(default=None)          # [sum n_pages] physical ids
    spare: np.ndarray = field(default=None)         # [SPARE_PAGES] physical ids
    num_blocks: int = 0
    width: int = 0
    block_table: np.ndarray = field(default=None)   # [R, width] int32
    q_codes: np.ndarray = field(default=None)       # [T, H, 128] uint8 (E4M3) or uint16 (bf16)
    q_dtype: str = "e4m3"

    @property
    def Rd(self):
        return len(self.dec_seq_lens)

    @property
    def Rp(self):
        return len(self.pre_ctx)

    @property
    def n_decode_rows(self):
        return self.Rd * self.query_len

    @property
    def n_prefill_rows(self):
        return int(self.pre_new.sum())

    @property
    def T(self):
        return self.n_decode_rows + self.n_prefill_rows

    @property
    def cu_seqlens_q(self):
        return np.concatenate([[0], np.cumsum(self.pre_new)]).astype(np.int32)

    def slots(self, r):
        """Physical slots (page * 128 + offset) of request r's tokens."""
        pos = np.arange(int(self.seq_lens[r]), dtype=np.int64)
        pg = self.phys[self.page_off[r] + pos // PAGE_TOKENS].astype(np.int64)
        return pg * PAGE_TOKENS + pos % PAGE_TOKENS

    def k_rows(self, r):
        """fp32 K rows [seq_len, 128] of request r (positions 0..seq_len-1)."""
        n = int(self.seq_lens[r])
        k = np.random.default_rng([self.seed, 1, r]).standard_normal(
            (n, HEAD_DIM), dtype=np.float32)
        if self.planted and r < self.Rd and n > 0:
            self._plant(r, k)
        return k

    def _plant(self, r, k):
        import torch
        hist = max((int(self.seq_lens[r]) - 1) // PAGE_TOKENS, 0)
        if hist == 0:
            return
        rng = np.random.default_rng([self.seed, 4, r])
        n_pl = max(1, int(round(self.planted * hist)))
        pages = rng.choice(hist, size=n_pl, replace=False)
        toks = rng.integers(0, PAGE_TOKENS, size=n_pl)
        rows = np.ascontiguousarray(self.q_codes[r * self.query_len:(r + 1) * self.query_len])
        if self.q_dtype == "bf16":
            qv = torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16).float().numpy()
        else:
            qv = torch.from_numpy(rows).view(torch.float8_e4m3fn).float().numpy()
        qv = qv.reshape(-1, HEAD_DIM)
        norms = np.linalg.norm(qv, axis=1, keepdims=True)
        unit = qv / np.where(norms > 0, norms, 1.0)
        direction = 3.0 * np.sign(unit.sum(axis=0))
        for pg, t in zip(pages, toks):
            k[pg * PAGE_TOKENS + t] += direction.astype(np.float32)

    def planted_pages(self, r):
        """Logical ids of the planted pages of decode request r."""
        hist = max((int(self.seq_lens[r]) - 1) // PAGE_TOKENS, 0)
        if not self.planted or hist == 0:
            return np.zeros(0, dtype=np.int64)
        rng = np.random.default_rng([self.seed, 4, r])
        n_pl = max(1, int(round(self.planted * hist)))
        return np.sort(rng.choice(hist, size=n_pl, replace=False))

    def request_slice(self, r):
        """Rows of the [T, H, 16] output owned by request r."""
        if r < self.Rd:
            return slice(r * self.query_len, (r + 1) * self.query_len)
        cu = self.cu_seqlens_q
        p = r - self.Rd
        return slice(self.n_decode_rows + int(cu[p]), self.n_decode_rows + int(cu[p + 1]))

    def poisoned_pool(self):
        """Host pool [num_blocks, 8704] uint8 filled with poison pages."""
        return np.tile(poison_page(), (self.num_blocks, 1))


def make_workload(name, seed=0, q_dtype="e4m3", **overrides):
    """The named workload; ``q_dtype`` "e4m3" (bytes) or "bf16" (bfloat16 bit
    patterns as uint16) for the index-Q, cast by torch from the same fp32
    draw either way."""
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    rng = np.random.default_rng([seed, 0])
    H = int(cfg["H"])
    dec = cfg.get("decode")
    pre = cfg.get("prefill")
    if dec is not None:
        if "seq_lens" in dec:
            dsl = np.asarray(dec["seq_lens"], dtype=np.int32)
        else:
            dsl = rng.integers(dec["lo"], dec["hi"], size=dec["R"], endpoint=True).astype(np.int32)
        ql = int(dec["query_len"])
    else:
        dsl = np.zeros(0, dtype=np.int32)
        ql = 0
    if pre is not None:
        if "ctx" in pre:
            ctx = np.asarray(pre["ctx"], dtype=np.int32)
            new = np.asarray(pre["new"], dtype=np.int32)
        else:
            ctx = rng.integers(pre["ctx_lo"], pre["ctx_hi"], size=pre["R"],
                               endpoint=True).astype(np.int32)
            new = np.full(pre["R"], pre["new"], dtype=np.int32)
    else:
        ctx = np.zeros(0, dtype=np.int32)
        new = np.zeros(0, dtype=np.int32)
    w = Workload(name=name, seed=seed, H=H, query_len=ql, dec_seq_lens=dsl,
                 pre_ctx=ctx, pre_new=new, planted=float(cfg.get("planted", 0.0)),
                 budget=cfg.get("budget"))
    w.seq_lens = np.concatenate([dsl, ctx + new]).astype(np.int32)
    w.n_pages = (-(-w.seq_lens.astype(np.int64) // PAGE_TOKENS)).astype(np.int64)
    w.page_off = np.concatenate([[0], np.cumsum(w.n_pages)[:-1]]).astype(np.int64)
    used = int(w.n_pages.sum())
    w.num_blocks = used + SPARE_PAGES
    perm = np.random.default_rng([seed, 3]).permutation(w.num_blocks).astype(np.int32)
    w.phys = perm[:used]
    w.spare = perm[used:]
    w.width = int(max(int(w.n_pages.max()) if len(w.n_pages) else 1, 1)) + 2
    R = len(w.seq_lens)
    w.block_table = np.full((R, w.width), w.spare[0], dtype=np.int32)
    for r in range(R):
        n = int(w.n_pages[r])
        w.block_table[r, :n] = w.phys[w.page_off[r]:w.page_off[r] + n]
    import torch
    qf = np.random.default_rng([seed, 2]).standard_normal((w.T, H, HEAD_DIM), dtype=np.float32)
    if q_dtype == "e4m3":
        w.q_codes = torch.from_numpy(qf).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    elif q_dtype == "bf16":
        w.q_codes = torch.from_numpy(qf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    else:
        raise ValueError(f"unknown index-Q dtype {q_dtype!r}")
    w.q_dtype = q_dtype
    return w


def host_pool(w, writer):
    """The whole pool on the host: poison, then every request's K rows stored
    by ``writer(pages, slots, k_rows)`` (the oracle's encoder in tests)."""
    pool = w.poisoned_pool()
    for r in range(len(w.seq_lens)):
        writer(pool, w.slots(r), w.k_rows(r))
    return pool
