"""Moves a seeded workload onto the device.

Uploads what the generator drew (fp32 K rows, E4M3 Q bytes, block table and
lengths) and asks the caller-supplied page writer (the library's
``mi_idx_insert_mxfp4``) to store K into a poisoned device pool.  No
arithmetic of the method lives here.
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from . import PAGE_BYTES, poison_page


class DeviceWorkload:
    """Device tensors of one workload: pool, q, block table, lengths."""

    def __init__(self, w, insert_fn, device="cuda", threads=16, pool_copies=1):
        self.w = w
        dev = torch.device(device)
        self.device = dev
        poison = torch.from_numpy(poison_page()).to(dev)
        self.pools = []
        for _ in range(pool_copies):
            pool = poison.repeat(w.num_blocks).view(w.num_blocks, PAGE_BYTES)
            self.pools.append(pool)
        self.pool = self.pools[0]
        R = len(w.seq_lens)
        batch = max(threads, 1) * 2
        with ThreadPoolExecutor(max_workers=max(threads, 1)) as ex:
            for b0 in range(0, R, batch):
                rs = list(range(b0, min(R, b0 + batch)))
                ks = list(ex.map(w.k_rows, rs))
                for r, k in zip(rs, ks):
                    if k.shape[0] == 0:
                        continue
                    kd = torch.from_numpy(k).to(dev)
                    sd = torch.from_numpy(w.slots(r)).to(dev)
                    for pool in self.pools:
                        insert_fn(kd, sd, pool)
                    del kd, sd
        if w.q_dtype == "bf16":
            self.q = torch.from_numpy(np.ascontiguousarray(w.q_codes).view(np.int16)).view(
                torch.bfloat16).to(dev)
        else:
            self.q = torch.from_numpy(np.ascontiguousarray(w.q_codes)).to(dev)
        self.block_table = torch.from_numpy(w.block_table).to(dev)
        self.seq_lens = torch.from_numpy(w.seq_lens).to(dev)
        self.Rd = w.Rd
        self.nd = w.n_decode_rows
        self.q_dec = self.q[:self.nd]
        self.q_pre = self.q[self.nd:]
        self.bt_dec = self.block_table[:w.Rd]
        self.bt_pre = self.block_table[w.Rd:]
        self.sl_dec = self.seq_lens[:w.Rd]
        self.sl_pre = self.seq_lens[w.Rd:]
        self.cu = torch.from_numpy(w.cu_seqlens_q).to(dev)
        self.ctx = torch.from_numpy(w.pre_ctx.astype(np.int32)).to(dev)
        self.out = torch.empty((w.T, w.H, 16), dtype=torch.int32, device=dev)

    def host_pool(self, i=0):
        return self.pools[i].cpu().numpy()
