"""The measurement probes of libmi_idx_probe.so on the GPU (small, fast
runs): each returns success, the CU count, clocks and the shader clock the
MFMA probe measures under load are plausible, and none writes its sink for
these inputs (the sink is written only for a value the caller never
passes)."""

import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_block_mxfp4_amd", "libmi_idx_probe.so"))
    vp, i64, ci, cu = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32
    lib.mi_idx_probe_read_stream.argtypes = [vp, i64, ci, vp, i64, vp]
    lib.mi_idx_probe_read_pages.argtypes = [vp, i64, vp, i64, ci, vp, i64, vp]
    lib.mi_idx_probe_mfma.argtypes = [ci, ci, ci, ci, cu, cu, vp, i64, vp, vp]
    lib.mi_idx_probe_device.argtypes = [vp, vp, vp]
    return lib


def test_probes_run():
    print("[gpu-test] probes", flush=True)
    lib = _lib()
    cus, clk, wall = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    assert lib.mi_idx_probe_device(ctypes.byref(cus), ctypes.byref(clk), ctypes.byref(wall)) == 0
    assert cus.value > 0 and clk.value > 0 and wall.value > 0
    s = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(cus.value * 64 * 256, dtype=torch.int32, device="cuda")
    buf = torch.ones(64 << 20, dtype=torch.uint8, device="cuda")
    assert lib.mi_idx_probe_read_stream(buf.data_ptr(), buf.numel(), 8, sink.data_ptr(),
                                        sink.numel(), s) == 0
    npages = buf.numel() // 8704
    order = torch.randperm(npages, dtype=torch.int32, device="cuda")
    assert lib.mi_idx_probe_read_pages(buf.data_ptr(), npages, order.data_ptr(), npages, 4,
                                       sink.data_ptr(), sink.numel(), s) == 0
    clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
    for kind in (0, 1):
        for fold in (0, 1):
            assert lib.mi_idx_probe_mfma(kind, fold, 64, 2, 0x22222222, 0x38383838,
                                         sink.data_ptr(), sink.numel(), clocks.data_ptr(), s) == 0
            torch.cuda.synchronize()
            shader, wall_ticks = (int(x) for x in clocks.cpu())
            assert shader > 0 and wall_ticks > 0
            mhz = shader / (wall_ticks / (wall.value * 1e3)) / 1e6
            assert 100 < mhz < 5000, mhz
    # the probes never write their sink for these operands
    assert int(sink.abs().sum().item()) == 0
