"""Benchmark of the MXFP4 lightning indexer hot path on one MI355X.

One step = one pass of the whole hot path over the mixed-step workload
(32 decode requests x 2 queries at 196608..262144 tokens, plus 2 prefill
chunks of 8192 rows over 131072-token histories, 4 index heads): the decode
plan (device kernel), the decode scorer, the prefill plan (host tiles + one
pinned H2D copy) and the prefill scorer, all writing one [16448, 4, 16] int32
buffer.  Inputs are resident in HBM before the timed region.  The decode phase
reads two pool copies in turn so the 0.5 GB of pages are not served from the
256 MB Infinity Cache.

Prints ONE JSON line.  Kernel times come from HIP events recorded on the
stream the kernels run on, inside the timed steps.  The CPU baseline is the
oracle timed on a bounded sample of the same workload on this host.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, GB/s
PEAK_FP8_TFLOPS = 5000.0        # dense FP8 MFMA (the FP8 x FP4 scaled MFMA runs at this rate)
METRIC = "index-K GB/s + query-rows/s (decode, prefill), % of HBM/MFMA peak, 1 GPU"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="mixed_step")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--pool-copies", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy three times (the reference "
                        "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return p.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def algorithmic(w):
    """Algorithmic work per step: decode index-K bytes (pages + block-table
    entries + Q + output) and prefill flops (2*128*128 per row, head and
    history page)."""
    dec_hist = np.maximum((w.dec_seq_lens.astype(np.int64) - 1) // 128, 0)
    nd = w.n_decode_rows
    dec_bytes = int(dec_hist.sum()) * (8704 + 4) + nd * w.H * (128 + 64)
    dec_pages = int(dec_hist.sum())
    cu = w.cu_seqlens_q
    pre_L = np.concatenate([(int(w.pre_ctx[r]) + np.arange(int(w.pre_new[r]))) // 128
                            for r in range(w.Rp)]) if w.Rp else np.zeros(0, dtype=np.int64)
    pre_flops = int(pre_L.sum()) * w.H * 2 * 128 * 128
    pre_pages = int(sum(max((int(w.seq_lens[w.Rd + r]) - 1) // 128, 0) for r in range(w.Rp)))
    pre_bytes = pre_pages * 8704 + w.n_prefill_rows * w.H * (128 + 64)
    return dict(dec_bytes=dec_bytes, dec_pages=dec_pages, pre_flops=pre_flops,
                pre_bytes=pre_bytes, pre_pages=pre_pages)


def measured_traffic(kernel, source):
    """HBM bytes per launch of `kernel` (FETCH_SIZE + WRITE_SIZE, scaled by the
    copy calibration) from the committed rocprofv3 summary, or None when the
    kernel's source has changed since the counters were taken."""
    import hashlib
    summary = os.path.join(ROOT, "profiles", "mixed_step_kernels.txt")
    src = os.path.join(ROOT, "sparse_attention_block_mxfp4_amd", "csrc", source)
    if not (os.path.exists(summary) and os.path.exists(src)):
        return None
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    for line in open(summary):
        f = line.split()
        if len(f) == 4 and f[0] == kernel and f[3] == digest:
            return int(float(f[1]) + float(f[2]))
    return None


def cpu_baseline(w):
    """The oracle on a bounded sample: two whole decode requests and 512 rows
    of one prefill request, scoring + selection only (pages encoded before
    the clock starts).  Extrapolated to the step by counts of requests and
    rows."""
    import oracle
    from threadpoolctl import threadpool_info

    cores = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])

    def request_pages(r):
        k = w.k_rows(r)
        pages = w.poisoned_pool()[:int(w.n_pages[r])].copy()
        oracle.write_pages(pages, np.arange(k.shape[0]), k)
        return pages

    est = 0.0
    sample_s = 0.0
    parts = []
    if w.Rd:
        nreq = min(2, w.Rd)
        t = 0.0
        for r in range(nreq):
            pages = request_pages(r)
            t0 = time.perf_counter()
            bt = np.arange(pages.shape[0], dtype=np.int32)[None, :]
            oracle.oracle_decode(w.q_codes[r * w.query_len:(r + 1) * w.query_len], pages, bt,
                                 w.dec_seq_lens[r:r + 1], w.query_len)
            t += time.perf_counter() - t0
        sample_s += t
        est += t / nreq * w.Rd
        parts.append(f"decode requests 0..{nreq - 1} ({w.query_len} rows x {w.H} heads each)")
    if w.Rp:
        r = w.Rd
        pages = request_pages(r)
        n = min(512, int(w.pre_new[0]))
        rows = np.arange(n)
        pos = int(w.pre_ctx[0]) + rows
        hist = int(pos.max() // 128)
        T0 = w.n_decode_rows
        t0 = time.perf_counter()
        kp = oracle.decode_pages(pages[:hist])
        t_pages = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.index_rows(oracle.e4m3fn_to_float(w.q_codes[T0:T0 + n]), pos, kp, 1.0)
        t_rows = time.perf_counter() - t0
        sample_s += t_pages + t_rows
        est += w.Rp * t_pages + t_rows * (w.n_prefill_rows / n)
        parts.append(f"prefill request {r}: page decode + {n} of {int(w.pre_new[0])} rows "
                     f"x {w.H} heads over {hist} pages")
    return {"value": w.T / est if est > 0 else None, "unit": "query rows/s", "cores": int(cores),
            "kind": "oracle", "sample": "; ".join(parts) +
            f"; {sample_s:.1f} s of oracle time, extrapolated to the step by request and row "
            f"counts (est. {est:.1f} s per step)",
            "cpu": _cpu_model()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {a.gpus} is not supported by this build "
              "(the multi-GPU sharding is described in DESIGN.md, not implemented).",
              file=sys.stderr)
        sys.exit(2)
    if a.copy_calibration:
        copy_calibration()
        return
    import torch

    import sparse_attention_block_mxfp4_amd as m
    import workloads as W
    from sparse_attention_block_mxfp4_amd.step import IndexerStep
    from workloads.device import DeviceWorkload

    torch.cuda.set_device(0)
    w = W.make_workload(a.workload, a.seed)
    print(f"[bench] staging {a.workload}: T={w.T} H={w.H} pages={w.num_blocks} "
          f"x{a.pool_copies} copies", file=sys.stderr, flush=True)
    dw = DeviceWorkload(w, m.mi_idx_insert_mxfp4, pool_copies=a.pool_copies)
    step = IndexerStep(w.H, w.width, max_decode_reqs=w.Rd, query_len=max(w.query_len, 1),
                       max_prefill_reqs=w.Rp, max_prefill_rows=w.n_prefill_rows)
    pre_cu = w.cu_seqlens_q
    pre_sl = w.seq_lens[w.Rd:]
    budget = w.budget or 0
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = []

    def one_step(i, record):
        pool = dw.pools[i % len(dw.pools)]
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if record else None
        if record:
            e[0].record(stream)
        step.plan(dw.sl_dec if w.Rd else None, pre_cu if w.Rp else None,
                  pre_sl if w.Rp else None, gather_budget_pages=budget)
        if record:
            e[1].record(stream)
        if w.Rd:
            step.decode(dw.q_dec, pool, dw.bt_dec, dw.sl_dec, dw.out[:dw.nd])
        if record:
            e[2].record(stream)
        if w.Rp:
            step.prefill(dw.q_pre, pool, dw.bt_pre, dw.cu, dw.sl_pre, dw.ctx, dw.out[dw.nd:])
        if record:
            e[3].record(stream)
            ev.append(e)

    for i in range(a.warmup):
        one_step(i, False)
    torch.cuda.synchronize()
    print(f"[bench] warmup done; timing {a.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(a.steps):
        one_step(i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    plan_ms = np.mean([e[0].elapsed_time(e[1]) for e in ev])
    dec_ms = np.mean([e[1].elapsed_time(e[2]) for e in ev])
    pre_ms = np.mean([e[2].elapsed_time(e[3]) for e in ev])
    ms_per_step = wall * 1e3 / a.steps
    alg = algorithmic(w)
    dec_gbps = alg["dec_bytes"] / (dec_ms * 1e-3) / 1e9 if w.Rd else 0.0
    pre_tflops = alg["pre_flops"] / (pre_ms * 1e-3) / 1e12 if w.Rp else 0.0
    phases = {
        "plan_ms": round(float(plan_ms), 4),
        "decode": {"kernel_ms": round(float(dec_ms), 4), "rows": w.n_decode_rows,
                   "pages": alg["dec_pages"], "algorithmic_bytes": alg["dec_bytes"],
                   "index_k_GBps": round(dec_gbps, 1),
                   "hbm_frac": round(dec_gbps / PEAK_HBM_GBPS, 4),
                   "rows_per_s": round(w.n_decode_rows / (dec_ms * 1e-3), 1) if w.Rd else None},
        "prefill": {"kernel_ms": round(float(pre_ms), 4), "rows": w.n_prefill_rows,
                    "pages": alg["pre_pages"], "algorithmic_flops": alg["pre_flops"],
                    "index_k_GBps": round(alg["pre_bytes"] / (pre_ms * 1e-3) / 1e9, 1)
                    if w.Rp else None,
                    "tflops": round(pre_tflops, 1),
                    "mfma_frac": round(pre_tflops / PEAK_FP8_TFLOPS, 4),
                    "rows_per_s": round(w.n_prefill_rows / (pre_ms * 1e-3), 1) if w.Rp else None},
    }
    roof_dec = {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(dec_gbps / PEAK_HBM_GBPS, 4),
                "traffic": measured_traffic("decode_score_kernel", "decode.hip"),
                "kernel": "decode_score_kernel + decode_merge_kernel"}
    roof_pre = {"bound": "mfma", "achieved": round(pre_tflops, 1), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(pre_tflops / PEAK_FP8_TFLOPS, 4),
                "traffic": measured_traffic("prefill_score_kernel", "prefill.hip"),
                "kernel": "prefill_score_kernel"}
    dominant = roof_pre if (w.Rp and pre_ms >= dec_ms) else roof_dec
    res = {
        "metric": METRIC,
        "value": round(w.T / (ms_per_step * 1e-3), 1),
        "unit": "query rows/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x fp4e2m1 (e8m0 scales) -> f32",
        "data": "synthetic",
        "config": {"workload": a.workload, "seed": a.seed, "T": w.T, "heads": w.H,
                   "decode_requests": w.Rd, "query_len": w.query_len,
                   "prefill_requests": w.Rp, "prefill_rows": w.n_prefill_rows,
                   "pool_pages": w.num_blocks, "pool_copies": a.pool_copies},
        "phases": phases,
        "roofline": dominant,
        "roofline_kernels": {"decode": roof_dec, "prefill": roof_pre},
    }
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
