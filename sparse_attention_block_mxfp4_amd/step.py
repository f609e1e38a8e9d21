"""One indexer step on the device: decode rows first, then prefill rows, into
one shared [T, H, 16] int32 buffer of logical page ids.

The split mirrors the vllm pages (``indexer_nvfp4`` MiniMaxM3IndexerNvfp4Impl
.forward and ``indexer_mxfp4`` MiniMaxM3IndexerRocmMxfp4Impl.forward: decode
rows occupy the first rows of the shared buffer, prefill rows follow; the
plans are built once per step, the scorers run once per layer).  The persistent
buffers (decode plan and workspace, prefill plan, workspace and pinned
staging) are allocated once for the maxima given to the constructor and
refilled in place every step, so a captured decode phase keeps valid
addresses.

Every call goes through the C ABI (``mi_idx_*``); this class only owns the
buffers.
"""

import collections

import torch

from . import (
    mi_idx_decode_plan_bytes,
    mi_idx_decode_workspace_bytes,
    mi_idx_plan_decode,
    mi_idx_plan_prefill,
    mi_idx_prefill_plan_bytes,
    mi_idx_prefill_workspace_bytes,
    mi_idx_score_topk_decode,
    mi_idx_score_topk_prefill,
)


# Pinned staging buffers of the prefill plan, used in turn, and how often a
# step records an event after its upload.  An event recorded on the stream
# leaves the GPU idle for a few microseconds between the kernels around it,
# so not every step records one: an event covers every upload enqueued before
# it, and a buffer is rewritten only NSTAGE plans after its last use, by
# which time an event at or after that use exists (GUARD_EVERY < NSTAGE).
NSTAGE = 16
GUARD_EVERY = 8


class IndexerStep:
    def __init__(self, num_heads, max_pages, max_decode_reqs=0, query_len=1,
                 max_prefill_reqs=0, max_prefill_rows=0, device="cuda"):
        self.H = int(num_heads)
        self.max_pages = int(max_pages)
        self.query_len = int(query_len)
        self.device = torch.device(device)
        self.dec_plan = self.dec_ws = None
        if max_decode_reqs > 0:
            self.dec_plan = torch.empty(mi_idx_decode_plan_bytes(max_decode_reqs),
                                        dtype=torch.uint8, device=self.device)
            self.dec_ws = torch.empty(
                mi_idx_decode_workspace_bytes(max_decode_reqs, self.query_len, self.H),
                dtype=torch.uint8, device=self.device)
        self.pre_plan = self.pre_ws = None
        self.pre_staging = []
        self._plans = 0                       # prefill plans made so far
        self._guards = collections.deque()    # (plan number, event after its upload)
        self.pre_launch = None
        if max_prefill_reqs > 0:
            nb = mi_idx_prefill_plan_bytes(max_prefill_reqs, max_prefill_rows, self.H)
            self.pre_plan = torch.empty(nb, dtype=torch.uint8, device=self.device)
            self.pre_ws = torch.empty(mi_idx_prefill_workspace_bytes(), dtype=torch.uint8,
                                      device=self.device)
            self.pre_staging = [torch.empty(nb, dtype=torch.uint8, pin_memory=True)
                                for _ in range(NSTAGE)]

    def plan(self, decode_seq_lens=None, prefill_cu_seqlens_q_host=None,
             prefill_seq_lens_host=None, gather_budget_pages=0, stream=None):
        """decode_seq_lens: device int32 [Rd]; prefill lengths: host arrays."""
        if decode_seq_lens is not None and decode_seq_lens.numel() > 0:
            mi_idx_plan_decode(decode_seq_lens, self.query_len, self.H, self.max_pages,
                               self.dec_plan, self.dec_ws, stream=stream)
        self.pre_launch = None
        if prefill_cu_seqlens_q_host is not None and len(prefill_seq_lens_host) > 0:
            n = self._plans
            k = n % NSTAGE
            if n >= NSTAGE:
                # the upload that last read buffer k must have completed
                last = n - NSTAGE
                while self._guards[0][0] < last:
                    self._guards.popleft()
                self._guards[0][1].synchronize()
            self.pre_launch = mi_idx_plan_prefill(
                prefill_cu_seqlens_q_host, prefill_seq_lens_host, self.H, gather_budget_pages,
                self.pre_staging[k], self.pre_plan, stream=stream)
            if n % GUARD_EVERY == 0:
                ev = torch.cuda.Event()
                ev.record(torch.cuda.current_stream() if stream is None else stream)
                self._guards.append((n, ev))
            self._plans = n + 1

    def decode(self, q, pages, block_table, seq_lens, out, scale=1.0, scores_out=None,
               stream=None):
        mi_idx_score_topk_decode(q, pages, block_table, seq_lens, self.query_len,
                                 self.max_pages, self.dec_plan, self.dec_ws, out, scale=scale,
                                 scores_out=scores_out, stream=stream)

    def prefill(self, q, pages, block_table, cu_seqlens_q, seq_lens, context_lens, out,
                scale=1.0, scores_out=None, stream=None):
        if self.pre_launch is None or self.pre_launch.num_lists == 0:
            return
        mi_idx_score_topk_prefill(q, pages, block_table, cu_seqlens_q, seq_lens, context_lens,
                                  self.max_pages, self.pre_plan, self.pre_launch, self.pre_ws,
                                  out, scale=scale, scores_out=scores_out, stream=stream)
