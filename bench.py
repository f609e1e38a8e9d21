"""Benchmark of the MXFP4 lightning indexer hot path on one MI355X.

One step = one pass of the whole hot path over the mixed-step workload
(32 decode requests x 2 queries at 196608..262144 tokens, plus 2 prefill
chunks of 8192 rows over 131072-token histories, 4 index heads): the decode
plan (device kernel), the decode scorer, the prefill plan (host tiles + one
pinned H2D copy) and the prefill scorer, all writing one [16448, 4, 16] int32
buffer.  Inputs are resident in HBM before the timed region.  The steps read
pool copies in turn (two for the mixed step's 0.5 GB of pages, more for
smaller pools) so that pages are not served from the 256 MB Infinity Cache.

Prints ONE JSON line.  The timed steps carry no events (``ms_per_step``,
``value``); per-phase kernel times come from the same steps run again right
after, with fence-free HIP timing events recorded on the stream the kernels
run on.  The CPU baseline is the oracle timed on a bounded sample of the same
workload on this host.
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
PEAK_BF16_TFLOPS = 2500.0       # dense bf16 MFMA (the path of a bf16 index-Q)
PEAK_FP4_TFLOPS = 10100.0       # dense MXFP4 x MXFP4 (both operands FP4; quoted, not the bound)
METRIC = "index-K GB/s + query-rows/s (decode, prefill), % of HBM/MFMA peak, 1 GPU"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    # Warm-up runs at least this many untimed steps and in any case until
    # --warmup-seconds of back-to-back GPU work have passed: the GPU needs
    # ~0.1 s of sustained work to reach its steady clocks (with only a few
    # warm-up steps the timed steps ran ~10 % slow).
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--warmup-seconds", type=float, default=0.25)
    p.add_argument("--no-ceiling", action="store_true",
                   help="skip the HBM read and MFMA ceiling probes (libmi_idx_probe.so)")
    p.add_argument("--workload", default="mixed_step")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--pool-copies", type=int, default=None,
                   help="pool copies read in turn (default: enough that two Infinity Caches' "
                        "worth of other copies is read between two uses of one, 2..16)")
    p.add_argument("--q-dtype", choices=["e4m3", "bf16"], default="e4m3",
                   help="index-Q dtype (E4M3 is the configured workload; bf16 runs the "
                        "bf16-MFMA path)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy three times (the reference "
                        "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    p.add_argument("--summarize-profiles", metavar="DIR",
                   help="only turn the rocprofv3 CSV output under DIR (prof_trace, "
                        "prof_fetch, prof_write, prof_copyf, prof_copyw, prof_sq) into "
                        "profiles/<workload>_kernels.txt")
    p.add_argument("--cpu-seconds", type=float, default=18.0,
                   help="oracle time budget of the CPU baseline sample")
    p.add_argument("--insert", action="store_true",
                   help="also time the fused qk-norm / rotary / MXFP4 insert of the step's T "
                        "new index-K rows (fp32, RMS norm, rotary dim 64 neox), outside the "
                        "timed step; reported under phases.norm_rope_insert")
    p.add_argument("--general", metavar="TOPK,INIT,LOCAL",
                   help="also time the general selection path (score calls writing every "
                        "history page's score, mi_idx_score_local, mi_idx_select_topk) on the "
                        "step's rows, outside the timed step; reported under phases.general")
    p.add_argument("--forced", metavar="TOPK,INIT,LOCAL",
                   help="also time the general forced-block selection (mi_idx_select_forced) "
                        "on the step's output, outside the timed step; reported under "
                        "phases.select_forced")
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
    qb = 256 if w.q_dtype == "bf16" else 128
    dec_bytes = int(dec_hist.sum()) * (8704 + 4) + nd * w.H * (qb + 64)
    dec_pages = int(dec_hist.sum())
    cu = w.cu_seqlens_q
    pre_L = np.concatenate([(int(w.pre_ctx[r]) + np.arange(int(w.pre_new[r]))) // 128
                            for r in range(w.Rp)]) if w.Rp else np.zeros(0, dtype=np.int64)
    pre_flops = int(pre_L.sum()) * w.H * 2 * 128 * 128
    pre_pages = int(sum(max((int(w.seq_lens[w.Rd + r]) - 1) // 128, 0) for r in range(w.Rp)))
    pre_bytes = pre_pages * 8704 + w.n_prefill_rows * w.H * (qb + 64)
    return dict(dec_bytes=dec_bytes, dec_pages=dec_pages, pre_flops=pre_flops,
                pre_bytes=pre_bytes, pre_pages=pre_pages)


INFINITY_CACHE_BYTES = 256 << 20


def auto_pool_copies(pool_bytes):
    """Copies read in turn so that between two uses of one copy the others
    move at least twice the Infinity Cache: 1 + ceil(2 * 256 MB / pool),
    within 2..16."""
    need = 1 + -(-2 * INFINITY_CACHE_BYTES // max(int(pool_bytes), 1))
    return int(min(max(need, 2), 16))


def code_digest(text):
    """Digest of C++ source text with comments and whitespace removed: it
    changes when the code does, not when a comment does."""
    import hashlib
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256("".join(text.split()).encode()).hexdigest()[:16]


def source_digest(name):
    """code_digest of a kernel source followed by the header it includes."""
    csrc = os.path.join(ROOT, "sparse_attention_block_mxfp4_amd", "csrc")
    return code_digest("".join(open(os.path.join(csrc, f)).read() for f in (name, "common.h")))


def measured_traffic(kernels, source, workload="mixed_step"):
    """HBM bytes per launch of the named kernels together (FETCH_SIZE +
    WRITE_SIZE, scaled by the copy calibration) from the committed rocprofv3
    summary of the same workload, or None when there is none, when any of
    the kernels is missing there or when its source has changed since the
    counters were taken."""
    summary = os.path.join(ROOT, "profiles", f"{workload}_kernels.txt")
    src = os.path.join(ROOT, "sparse_attention_block_mxfp4_amd", "csrc", source)
    if not (os.path.exists(summary) and os.path.exists(src)):
        return None
    digest = source_digest(source)
    found = {}
    for line in open(summary):
        f = line.split()
        if len(f) == 4 and f[0] in kernels and f[3] == digest:
            found[f[0]] = float(f[1]) + float(f[2])
    if set(found) != set(kernels):
        return None
    return int(sum(found.values()))


class TimingEvent:
    """A HIP timing event created with hipEventDisableSystemFence.  Recording
    a default event performs a system-scope fence (caches written back and
    invalidated), which left the GPU idle for about 5 us between the kernels
    around it and inside every interval it opens; this one only timestamps.
    Created through the HIP runtime already loaded in the process (the same
    library path, so the same runtime as torch's streams).  Every loop below
    creates its events before it starts: creating one while the GPU is busy
    measured as slow as a device synchronisation."""
    _hip = None

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes
            path = next((line.split()[-1] for line in open("/proc/self/maps")
                         if "libamdhip64.so" in line), None)
            if path is None:
                raise RuntimeError("TimingEvent: the HIP runtime (libamdhip64.so) is not loaded "
                                   "in this process; initialise torch.cuda first")
            h = ctypes.CDLL(path)
            vp = ctypes.c_void_p
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            h.hipEventRecord.argtypes = [vp, vp]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            h.hipEventDestroy.argtypes = [vp]
            cls._hip = h
        return cls._hip

    FLAGS = 0x20000000   # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        self._ct = ctypes
        self.ev = ctypes.c_void_p()
        st = self._runtime().hipEventCreateWithFlags(ctypes.byref(self.ev), self.FLAGS)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")

    def record(self, stream):
        st = self._hip.hipEventRecord(self.ev, self._ct.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def elapsed_time(self, end):
        """Milliseconds from this event to ``end`` (both completed)."""
        ms = self._ct.c_float()
        st = self._hip.hipEventElapsedTime(self._ct.byref(ms), self.ev, end.ev)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


def hbm_ceilings(torch, reps=5):
    """Read ceilings of this GPU's HBM, for the decode phase to be reported
    against next to the 8 TB/s figure: a coalesced read of a 2 GiB buffer,
    and whole 8704-byte pages of a 1 GiB pool read in a random order (the
    decode's access pattern) with 2 pages per wave and with 28 (the decode
    plan's item length on the mixed step).  Median of ``reps`` launches
    each, HIP events on the launching stream."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_block_mxfp4_amd",
                                   "libmi_idx_probe.so"))
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.mi_idx_probe_read_stream.argtypes = [vp, i64, ctypes.c_int, vp, i64, vp]
    lib.mi_idx_probe_read_pages.argtypes = [vp, i64, vp, i64, ctypes.c_int, vp, i64, vp]
    stream = torch.cuda.current_stream()
    sink = torch.zeros(1 << 22, dtype=torch.int32, device="cuda")
    buf = torch.ones(2 << 30, dtype=torch.uint8, device="cuda")
    npages = (1 << 30) // 8704
    pool = buf[:npages * 8704]
    order = torch.from_numpy(np.random.default_rng(0).permutation(npages).astype(np.int32)).cuda()

    def timed(call, nbytes):
        ts = [(TimingEvent(), TimingEvent()) for _ in range(reps)]
        call()
        for e0, e1 in ts:
            e0.record(stream)
            st = call()
            e1.record(stream)
            if st != 0:
                raise RuntimeError(f"probe failed with status {st}")
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in ts]))
        return round(nbytes / (ms * 1e-3) / 1e9, 1)

    s = stream.cuda_stream
    # 8 workgroups per CU: within 1 % of the best of 1..16 on a 1-4 GiB sweep
    out = {"read_stream_GBps": timed(lambda: lib.mi_idx_probe_read_stream(
        buf.data_ptr(), buf.numel(), 8, sink.data_ptr(), sink.numel(), s), buf.numel())}
    for per_wave in (2, 28):
        out[f"random_pages_{per_wave}_per_wave_GBps"] = timed(
            lambda: lib.mi_idx_probe_read_pages(pool.data_ptr(), npages, order.data_ptr(),
                                                npages, per_wave, sink.data_ptr(), sink.numel(),
                                                s), npages * 8704)
    out["spec_GBps"] = PEAK_HBM_GBPS
    out["bytes"] = {"read_stream": int(buf.numel()), "random_pages": int(npages * 8704)}
    del buf, pool, order, sink
    torch.cuda.empty_cache()
    return out


def mfma_ceilings(torch, reps=5, iters=20000):
    """Matrix-core ceilings of this GPU, for the prefill phase to be reported
    against next to the dense specification figures: the scaled FP4 x FP8
    16x16x128 MFMA the scorer issues, and the bf16 16x16x32 MFMA of a
    bfloat16 query, each as 8 accumulating chains per wave (the instruction's
    rate) and as the scorer's zeroed-accumulator + max3-fold pipeline, with
    1 and 2 workgroups of 4 waves per compute unit (1 and 2 waves per SIMD).
    Median of ``reps`` launches each, HIP events on the launching stream; the
    shader clock under load is workgroup 0's shader-clock ticks over its
    wall-clock ticks."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_block_mxfp4_amd",
                                   "libmi_idx_probe.so"))
    vp, i64, ci, cu = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32
    lib.mi_idx_probe_mfma.argtypes = [ci, ci, ci, ci, cu, cu, vp, i64, vp, vp]
    cus, clk, wall = ci(), ci(), ci()
    if lib.mi_idx_probe_device(ctypes.byref(cus), ctypes.byref(clk), ctypes.byref(wall)) != 0:
        raise RuntimeError("mi_idx_probe_device failed")
    stream = torch.cuda.current_stream()
    sink = torch.zeros(cus.value * 2 * 256, dtype=torch.int32, device="cuda")
    clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
    out = {"compute_units": cus.value, "clock_MHz_reported": clk.value / 1e3}
    flops_per = {"scaled_fp4_fp8_16x16x128": 65536, "bf16_16x16x32": 16384}
    for kind, name in enumerate(flops_per):
        for fold, mode in ((0, "chains"), (1, "fold")):
            for bpc in (1, 2):
                def call():
                    st = lib.mi_idx_probe_mfma(kind, fold, iters, bpc, 0x22222222, 0x38383838,
                                               sink.data_ptr(), sink.numel(),
                                               clocks.data_ptr(), stream.cuda_stream)
                    if st != 0:
                        raise RuntimeError(f"mi_idx_probe_mfma failed with status {st}")
                ts = [(TimingEvent(), TimingEvent()) for _ in range(reps)]
                call()
                for e0, e1 in ts:
                    e0.record(stream)
                    call()
                    e1.record(stream)
                torch.cuda.synchronize()
                ms = float(np.median([x.elapsed_time(y) for x, y in ts]))
                flops = cus.value * bpc * 4 * iters * 8 * flops_per[name]
                out[f"{name}_{mode}_{bpc}_waves_per_simd_TFLOPs"] = round(
                    flops / (ms * 1e-3) / 1e12, 1)
                if kind == 0 and fold == 0 and bpc == 2:
                    shader, wall_ticks = (int(x) for x in clocks.cpu())
                    out["clock_MHz_under_mfma_load"] = round(
                        shader / (wall_ticks / (wall.value * 1e3)) / 1e6, 1)
    out["spec_TFLOPs"] = {"fp8": PEAK_FP8_TFLOPS, "bf16": PEAK_BF16_TFLOPS}
    del sink, clocks
    return out


def cpu_baseline(w, budget_s):
    """The oracle on a bounded sample of the step: whole decode requests
    (scoring + selection) until about a third of the time budget is spent,
    then blocks of 256 rows of the first prefill request until the rest is;
    pages are encoded before the clock starts.  Extrapolated to the step by
    the count of decode requests, and for prefill by the history pages
    decoded and the (row, page) pairs scored.  BLAS runs one thread per core
    this process may use (its CPU affinity)."""
    from threadpoolctl import threadpool_limits
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(cores):
        return _cpu_baseline(w, budget_s, cores)


def _cpu_baseline(w, budget_s, cores):
    import oracle
    from threadpoolctl import threadpool_info

    blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])

    def request_pages(r):
        k = w.k_rows(r)
        pages = w.poisoned_pool()[:int(w.n_pages[r])].copy()
        oracle.write_pages(pages, np.arange(k.shape[0]), k)
        return pages

    est = 0.0
    sample_s = 0.0
    parts = []
    if w.Rd:
        t, nreq = 0.0, 0
        dec_budget = budget_s / 3 if w.Rp else budget_s
        while nreq < w.Rd and t < dec_budget:
            pages = request_pages(nreq)
            t0 = time.perf_counter()
            bt = np.arange(pages.shape[0], dtype=np.int32)[None, :]
            oracle.oracle_decode(w.q_codes[nreq * w.query_len:(nreq + 1) * w.query_len], pages,
                                 bt, w.dec_seq_lens[nreq:nreq + 1], w.query_len,
                                 q_dtype=w.q_dtype)
            t += time.perf_counter() - t0
            nreq += 1
        sample_s += t
        est += t / nreq * w.Rd
        parts.append(f"decode requests 0..{nreq - 1} of {w.Rd} ({w.query_len} rows x {w.H} "
                     f"heads each)")
    if w.Rp:
        r = w.Rd
        pages = request_pages(r)
        new = int(w.pre_new[0])
        T0 = w.n_decode_rows
        pos_all = int(w.pre_ctx[0]) + np.arange(new)
        t0 = time.perf_counter()
        kp = oracle.decode_pages(pages[:int(pos_all.max() // 128)])
        t_pages = time.perf_counter() - t0
        t_rows, n = 0.0, 0
        while n < new and t_pages + t_rows < budget_s - sample_s:
            m = min(256, new - n)
            t0 = time.perf_counter()
            oracle.index_rows(oracle.q_values(w.q_codes[T0 + n:T0 + n + m], w.q_dtype),
                              pos_all[n:n + m], kp, 1.0)
            t_rows += time.perf_counter() - t0
            n += m
        sample_s += t_pages + t_rows
        # Extrapolated by work, not counts, since requests differ in length:
        # page decoding by the history pages a request's rows reach, scoring
        # by (row, page) pairs (a row scores its p // 128 history pages and
        # its local page).
        hist = [(int(c) + int(q) - 1) // 128 if q > 0 else 0 for c, q in zip(w.pre_ctx, w.pre_new)]
        row_pages = sum(int(np.sum((int(c) + np.arange(int(q))) // 128 + 1))
                        for c, q in zip(w.pre_ctx, w.pre_new))
        est += (t_pages * sum(hist) / max(hist[0], 1)
                + t_rows * row_pages / max(int(np.sum(pos_all[:n] // 128 + 1)), 1))
        parts.append(f"prefill request {r}: page decode + rows 0..{n - 1} of {new} x {w.H} "
                     f"heads over up to {int(pos_all[n - 1] // 128)} pages")
    return {"value": w.T / est if est > 0 else None, "unit": "query rows/s", "cores": int(cores),
            "kind": "oracle", "sample": "; ".join(parts) +
            f"; {sample_s:.1f} s of oracle time, extrapolated to the step by decode requests "
            f"and by prefill pages and (row, page) pairs (est. {est:.1f} s per step)",
            "sample_seconds": round(sample_s, 4), "step_seconds_est": round(est, 4),
            "blas_threads": int(blas_threads), "affinity_cpus": int(cores),
            "host_cpus": os.cpu_count(), "cpu": _cpu_model()}


def _cpu_model():
    """The host CPU as /proc/cpuinfo names it (model, family/model/stepping,
    MHz)."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (x.strip() for x in line.split(":", 1))
                if k in ("model name", "cpu family", "model", "stepping", "cpu MHz") and \
                        k not in info:
                    info[k] = v
            if not line.strip() and info:
                break
    except OSError:
        pass
    if not info:
        return "unknown"
    return (f"{info.get('model name', 'unknown')} (family {info.get('cpu family', '?')}, "
            f"model {info.get('model', '?')}, stepping {info.get('stepping', '?')}, "
            f"{info.get('cpu MHz', '?')} MHz)")


KERNEL_SOURCES = {"decode_plan_kernel": "decode.hip", "decode_score_kernel": "decode.hip",
                  "decode_merge_kernel": "decode.hip", "prefill_score_kernel": "prefill.hip",
                  "prefill_merge_kernel": "prefill.hip", "insert_kernel": "insert.hip"}
def profile_commands(workload):
    """The rocprofv3 runs behind profiles/<workload>_kernels.txt (W = the
    workload option, empty for the default mixed step).  Counter passes run
    two steps after one warm-up step (no time-bounded warm-up), without the
    HBM-ceiling probes."""
    W = "" if workload == "mixed_step" else f" --workload {workload}"
    short = f"--steps 2 --warmup 1 --warmup-seconds 0 --no-cpu-baseline --no-ceiling{W}"
    return [
        ("kernel trace + stats (the bench's own timed configuration)",
         "rocprofv3 --kernel-trace --stats -T -f csv -d DIR/prof_trace -o trace"
         f" -- python bench.py --no-cpu-baseline --no-ceiling{W}"),
        ("FETCH_SIZE", "rocprofv3 --pmc FETCH_SIZE -T -f csv -d DIR/prof_fetch -o fetch"
         f" -- python bench.py {short}"),
        ("WRITE_SIZE", "rocprofv3 --pmc WRITE_SIZE -T -f csv -d DIR/prof_write -o write"
         f" -- python bench.py {short}"),
        ("copy calibration, FETCH_SIZE", "rocprofv3 --pmc FETCH_SIZE -T -f csv -d DIR/prof_copyf"
         " -o copyf -- python bench.py --copy-calibration"),
        ("copy calibration, WRITE_SIZE", "rocprofv3 --pmc WRITE_SIZE -T -f csv -d DIR/prof_copyw"
         " -o copyw -- python bench.py --copy-calibration"),
        ("SQ counters", "rocprofv3 --pmc SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS "
         "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVE_CYCLES GRBM_GUI_ACTIVE -T -f csv "
         f"-d DIR/prof_sq -o sq -- python bench.py {short}"),
        ("summary", f"python bench.py --summarize-profiles DIR{W}"),
    ]


def summarize_profiles(d, workload):
    """Write profiles/<workload>_kernels.txt from the rocprofv3 CSVs under d."""
    import collections
    import csv

    def counters(path):
        out = collections.defaultdict(list)
        for row in csv.DictReader(open(path)):
            out[(row["Kernel_Name"], row["Counter_Name"])].append(float(row["Counter_Value"]))
        return out

    def per_kernel(cs, kernel, counter, part=False):
        vals = [v for (k, c), v in cs.items()
                if (kernel in k if part else k.startswith(kernel)) and c == counter]
        return sum(vals[0]) / len(vals[0]) if vals else None

    sha = source_digest

    stats = list(csv.DictReader(open(os.path.join(d, "prof_trace", "trace_kernel_stats.csv"))))
    fetch = counters(os.path.join(d, "prof_fetch", "fetch_counter_collection.csv"))
    write = counters(os.path.join(d, "prof_write", "write_counter_collection.csv"))
    cf = counters(os.path.join(d, "prof_copyf", "copyf_counter_collection.csv"))
    cw = counters(os.path.join(d, "prof_copyw", "copyw_counter_collection.csv"))
    copy_f = per_kernel(cf, "copyBuffer", "FETCH_SIZE", part=True)
    copy_w = per_kernel(cw, "copyBuffer", "WRITE_SIZE", part=True)
    gib = float(1 << 30)
    f_factor = gib / (copy_f * 1024)
    w_factor = gib / (copy_w * 1024)
    out = [f"# rocprofv3 summary: {workload} workload (bench.py defaults), one MI355X",
           "#", "# commands (run from the repository root; DIR = the output folder):"]
    for what, cmd in profile_commands(workload):
        out.append(f"#   {what}: {cmd}")
    out.append(f"# copy calibration: a plain 1 GiB device copy reads FETCH_SIZE {copy_f:.1f} KiB "
               f"(factor {f_factor:.4f}) and WRITE_SIZE {copy_w:.1f} KiB (factor {w_factor:.4f}) "
               "per launch")
    out += ["", "## kernel stats (insert_kernel stages the pools outside the timed steps)",
            "%-24s %6s %14s %14s %14s" % ("kernel", "calls", "avg_ns", "min_ns", "max_ns")]
    for row in stats:
        out.append("%-24s %6s %14.0f %14s %14s" % (row["Name"][:24], row["Calls"],
                                                   float(row["AverageNs"]), row["MinNs"],
                                                   row["MaxNs"]))
    out += ["", "## HBM traffic per launch (counter KiB x 1024 x calibration factor)",
            "%-24s %16s %16s %s" % ("kernel", "fetch_bytes", "write_bytes", "source_digest")]
    for k in ["decode_plan_kernel", "decode_score_kernel", "decode_merge_kernel",
              "prefill_score_kernel", "prefill_merge_kernel"]:
        fv, wv = per_kernel(fetch, k, "FETCH_SIZE"), per_kernel(write, k, "WRITE_SIZE")
        if fv is None or wv is None:
            continue
        out.append("%-24s %16.0f %16.0f %s" % (k, fv * 1024 * f_factor, wv * 1024 * w_factor,
                                               sha(KERNEL_SOURCES[k])))
    sq_path = os.path.join(d, "prof_sq", "sq_counter_collection.csv")
    if os.path.exists(sq_path):
        sq = counters(sq_path)
        out += ["", "## SQ counters per launch (GRBM_GUI_ACTIVE is summed over the 8 XCDs; "
                "MFMA busy is summed over the 1024 SIMDs)"]
        for k in ["prefill_score_kernel", "prefill_merge_kernel", "decode_score_kernel",
                  "decode_merge_kernel"]:
            g = per_kernel(sq, k, "GRBM_GUI_ACTIVE")
            if g is None:
                continue
            vals = {c: per_kernel(sq, k, c) for c in
                    ["SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS",
                     "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES"]}
            cyc = g / 8
            line = f"{k}: cycles {cyc:.0f}"
            for c, v in vals.items():
                line += f" {c[3:]} {v:.0f}"
            if vals["SQ_VALU_MFMA_BUSY_CYCLES"]:
                line += "  mfma_util %.1f%%" % (100 * vals["SQ_VALU_MFMA_BUSY_CYCLES"] /
                                                 (cyc * 1024))
            if vals["SQ_INSTS_MFMA"]:
                line += "  valu_per_mfma %.2f" % (vals["SQ_INSTS_VALU"] / vals["SQ_INSTS_MFMA"])
            out.append(line)
    path = os.path.join(ROOT, "profiles", f"{workload}_kernels.txt")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    open(path, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {a.gpus} is not supported: sharding over "
              "several GPUs (decode by pages with one all-gather of the partial lists, "
              "prefill by row tiles) is designed but not implemented.", file=sys.stderr)
        sys.exit(2)
    if a.copy_calibration:
        copy_calibration()
        return
    if a.summarize_profiles:
        summarize_profiles(a.summarize_profiles, a.workload)
        return
    import torch

    import sparse_attention_block_mxfp4_amd as m
    import workloads as W
    from sparse_attention_block_mxfp4_amd.step import IndexerStep
    from workloads.device import DeviceWorkload

    torch.cuda.set_device(0)
    w = W.make_workload(a.workload, a.seed, q_dtype=a.q_dtype)
    if a.pool_copies is None:
        a.pool_copies = auto_pool_copies(w.num_blocks * 8704)
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

    def one_step(i, e=None):
        pool = dw.pools[i % len(dw.pools)]
        record = e is not None
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

    tw = time.perf_counter()
    nwarm = 0
    while nwarm < a.warmup or time.perf_counter() - tw < a.warmup_seconds:
        for _ in range(10 if nwarm >= a.warmup else 1):
            one_step(nwarm)
            nwarm += 1
        if nwarm >= a.warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - tw
    print(f"[bench] warmup done ({nwarm} steps, {warm_s:.2f} s); timing {a.steps} steps",
          file=sys.stderr, flush=True)
    # The timed steps carry no events.  The per-phase kernel times come from
    # the same steps run again right after, with timing events (TimingEvent:
    # no system-scope fence) around each phase on the stream the kernels are
    # launched on.
    t0 = time.perf_counter()
    for i in range(a.steps):
        one_step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = [[TimingEvent() for _ in range(4)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(a.steps):
        one_step(i, ev[i])
    torch.cuda.synchronize()
    wall_instrumented = time.perf_counter() - t1

    plan_ms = np.mean([e[0].elapsed_time(e[1]) for e in ev])
    dec_ms = np.mean([e[1].elapsed_time(e[2]) for e in ev])
    pre_ms = np.mean([e[2].elapsed_time(e[3]) for e in ev])
    ms_per_step = wall * 1e3 / a.steps
    alg = algorithmic(w)
    dec_gbps = alg["dec_bytes"] / (dec_ms * 1e-3) / 1e9 if w.Rd else 0.0
    pre_tflops = alg["pre_flops"] / (pre_ms * 1e-3) / 1e12 if w.Rp else 0.0
    peak_mfma = PEAK_BF16_TFLOPS if w.q_dtype == "bf16" else PEAK_FP8_TFLOPS
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
                    "mfma_frac": round(pre_tflops / peak_mfma, 4),
                    "rows_per_s": round(w.n_prefill_rows / (pre_ms * 1e-3), 1) if w.Rp else None},
    }
    roof_dec = {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(dec_gbps / PEAK_HBM_GBPS, 4),
                "traffic": (measured_traffic(("decode_score_kernel", "decode_merge_kernel"),
                                             "decode.hip", a.workload)
                            if w.q_dtype == "e4m3" else None),
                "kernel": "decode_score_kernel + decode_merge_kernel"}
    # the prefill phase is the scorer and, when the plan split tiles, the merge
    pre_kernels = ("prefill_score_kernel",) + (
        ("prefill_merge_kernel",) if step.pre_launch is not None and step.pre_launch.num_merges
        else ())
    roof_pre = {"bound": "mfma", "achieved": round(pre_tflops, 1), "peak": peak_mfma,
                "unit": "TFLOP/s", "frac": round(pre_tflops / peak_mfma, 4),
                "traffic": (measured_traffic(pre_kernels, "prefill.hip", a.workload)
                            if w.q_dtype == "e4m3" else None),
                "kernel": " + ".join(pre_kernels)}
    if w.q_dtype == "e4m3":
        # the sheet's FP4 x FP4 figure, for reference: the E4M3 query operand
        # makes the instruction run at the FP8 rate, the bound used above
        roof_pre["mxfp4_sheet_peak"] = PEAK_FP4_TFLOPS
        roof_pre["frac_of_mxfp4_sheet"] = round(pre_tflops / PEAK_FP4_TFLOPS, 4)
    dominant = roof_pre if (w.Rp and pre_ms >= dec_ms) else roof_dec
    res = {
        "metric": METRIC,
        "value": round(w.T / (ms_per_step * 1e-3), 1),
        "unit": "query rows/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "warmup_run": {"steps": nwarm, "seconds": round(warm_s, 3)},
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_with_phase_events": round(wall_instrumented * 1e3 / a.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 x fp4e2m1 (e8m0 scales, converted to bf16) -> f32" if w.q_dtype == "bf16"
                  else "fp8e4m3 x fp4e2m1 (e8m0 scales) -> f32"),
        "data": "synthetic",
        "config": {"workload": a.workload, "seed": a.seed, "q_dtype": w.q_dtype, "T": w.T,
                   "heads": w.H,
                   "decode_requests": w.Rd, "query_len": w.query_len,
                   "prefill_requests": w.Rp, "prefill_rows": w.n_prefill_rows,
                   "pool_pages": w.num_blocks, "pool_copies": a.pool_copies},
        "phases": phases,
        "roofline": dominant,
        "roofline_kernels": {"decode": roof_dec, "prefill": roof_pre},
    }
    if a.insert:
        n_ins = w.T
        gen = torch.Generator(device="cuda").manual_seed(a.seed)
        k_new = torch.randn((n_ins, 128), device="cuda", generator=gen)
        wn = torch.rand(128, device="cuda", generator=gen) + 0.5
        pos_new = torch.randint(0, 1 << 20, (n_ins,), device="cuda", generator=gen)
        ins_pages = torch.zeros(((n_ins + 127) // 128) * 8704, dtype=torch.uint8, device="cuda")
        slot_new = torch.randperm(n_ins, device="cuda", generator=gen)
        call = lambda: m.mi_idx_norm_rope_insert_mxfp4(  # noqa: E731
            k_new, slot_new, ins_pages, norm_weight=wn, norm_eps=1e-6, positions=pos_new,
            rotary_dim=64, rope_base=10000.0, rope_style=0)
        times = [(TimingEvent(), TimingEvent()) for _ in range(50)]
        for _ in range(20):
            call()
        for e0, e1 in times:
            e0.record(stream)
            call()
            e1.record(stream)
        torch.cuda.synchronize()
        ins_ms = float(np.median([x.elapsed_time(y) for x, y in times]))
        ins_bytes = n_ins * (128 * 4 + 68 + 8 + 8)
        phases["norm_rope_insert"] = {
            "rows": n_ins, "rotary_dim": 64, "kernel_ms": round(ins_ms, 4),
            "algorithmic_bytes": ins_bytes,
            "GBps": round(ins_bytes / (ins_ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(ins_bytes / (ins_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
    if a.forced:
        topk, init, local = (int(x) for x in a.forced.split(","))
        max_k_tiles = -(-int(np.max(w.seq_lens)) // 128)
        sel_out = torch.empty((w.T, w.H, topk), dtype=torch.int32, device="cuda")
        times = [(TimingEvent(), TimingEvent()) for _ in range(50)]
        for _ in range(20):
            m.mi_idx_select_forced(dw.out, topk, init, local, max_k_tiles, out=sel_out)
        for e0, e1 in times:
            e0.record(stream)
            m.mi_idx_select_forced(dw.out, topk, init, local, max_k_tiles, out=sel_out)
            e1.record(stream)
        torch.cuda.synchronize()
        sel_ms = float(np.median([x.elapsed_time(y) for x, y in times]))
        sel_bytes = w.T * w.H * (16 + topk) * 4
        phases["select_forced"] = {
            "topk": topk, "init_blocks": init, "local_blocks": local,
            "max_k_tiles": max_k_tiles, "kernel_ms": round(sel_ms, 4),
            "algorithmic_bytes": sel_bytes,
            "GBps": round(sel_bytes / (sel_ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(sel_bytes / (sel_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
    if a.general:
        topk, init, local = (int(x) for x in a.general.split(","))
        max_k_tiles = -(-int(np.max(w.seq_lens)) // 128)
        loc = torch.empty((w.T, w.H), device="cuda")
        sel = torch.empty((w.T, w.H, topk), dtype=torch.int32, device="cuda")
        sc_all = torch.empty((w.T, w.H, w.width), device="cuda")
        pool = dw.pools[0]

        def gen_parts(e=None):
            record = e is not None
            if record:
                e[0].record(stream)
            step.plan(dw.sl_dec if w.Rd else None, pre_cu if w.Rp else None,
                      pre_sl if w.Rp else None, gather_budget_pages=budget)
            if w.Rd:
                step.decode(dw.q_dec, pool, dw.bt_dec, dw.sl_dec, dw.out[:dw.nd],
                            scores_out=sc_all[:dw.nd])
            if w.Rp:
                step.prefill(dw.q_pre, pool, dw.bt_pre, dw.cu, dw.sl_pre, dw.ctx, dw.out[dw.nd:],
                             scores_out=sc_all[dw.nd:])
            if record:
                e[1].record(stream)
            if w.Rd:
                m.mi_idx_score_local(dw.q_dec, pool, dw.bt_dec, w.width, local_out=loc[:dw.nd],
                                     seq_lens=dw.sl_dec, query_len=w.query_len)
            if w.Rp:
                m.mi_idx_score_local(dw.q_pre, pool, dw.bt_pre, w.width, local_out=loc[dw.nd:],
                                     cu_seqlens_q=dw.cu, context_lens=dw.ctx)
            if record:
                e[2].record(stream)
            m.mi_idx_select_topk(dw.out, sc_all, topk, init, local, max_k_tiles,
                                 local_scores=loc, out=sel)
            if record:
                e[3].record(stream)
            return e
        evs = [[TimingEvent() for _ in range(4)] for _ in range(10)]
        for _ in range(5):
            gen_parts()
        for e in evs:
            gen_parts(e)
        torch.cuda.synchronize()
        med = lambda i, j: float(np.median([x[i].elapsed_time(x[j]) for x in evs]))  # noqa: E731
        hist_rows = int(alg["pre_flops"] // (w.H * 2 * 128 * 128)) + int(
            sum(max(0, (int(sl) - w.query_len + i) // 128) for sl in w.dec_seq_lens
                for i in range(w.query_len)))
        phases["general"] = {
            "topk": topk, "init_blocks": init, "local_blocks": local, "max_k_tiles": max_k_tiles,
            "score_with_all_scores_ms": round(med(0, 1), 4),
            "local_scores_ms": round(med(1, 2), 4),
            "select_topk_ms": round(med(2, 3), 4),
            "rows_x_heads": w.T * w.H,
            "history_scores": hist_rows * w.H,
            "select_algorithmic_bytes": hist_rows * w.H * 4 + w.T * w.H * (64 + 4 + 4 * topk),
            "select_GBps": round((hist_rows * w.H * 4 + w.T * w.H * (64 + 4 + 4 * topk)) /
                                 (med(2, 3) * 1e-3) / 1e9, 1)}
    if not a.no_ceiling:
        print("[bench] HBM read ceilings", file=sys.stderr, flush=True)
        ceil = hbm_ceilings(torch)
        res["hbm_ceiling"] = ceil
        if w.Rd:
            roof_dec["frac_of_read_stream"] = round(dec_gbps / ceil["read_stream_GBps"], 4)
            roof_dec["frac_of_random_pages"] = round(
                dec_gbps / ceil["random_pages_2_per_wave_GBps"], 4)
        print("[bench] MFMA ceilings", file=sys.stderr, flush=True)
        mc = mfma_ceilings(torch)
        res["mfma_ceiling"] = mc
        if w.Rp:
            inst = "bf16_16x16x32" if w.q_dtype == "bf16" else "scaled_fp4_fp8_16x16x128"
            roof_pre["frac_of_instruction_rate"] = round(
                pre_tflops / mc[f"{inst}_chains_2_waves_per_simd_TFLOPs"], 4)
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
