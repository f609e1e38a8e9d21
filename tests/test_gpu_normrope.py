"""The fused qk-norm / rotary / MXFP4 insert on the GPU
(``mi_idx_norm_rope_insert_mxfp4``, through the C ABI) against the oracle's
fp64 norm and rotation (``oracle.norm_rope_rows``) and its MXFP4 encoder:
scale bytes and codes equal except where the exact value sits within 1e-5
of a rounding boundary (``tests/checker.compare_encoded``).  Without norm and
rotation the bytes equal the plain insert's exactly."""

import numpy as np
import pytest
import torch

import oracle
from tests import checker
from tests.gpu_common import lib

pytestmark = pytest.mark.gpu


def _rows(rng, n, dtype):
    k = (rng.standard_normal((n, 128)) * rng.uniform(0.01, 50, size=(n, 1))).astype(np.float32)
    kt = torch.from_numpy(k)
    if dtype == "bf16":
        kt = kt.to(torch.bfloat16)
    exact = kt.to(torch.float64).numpy()            # the values the kernel reads
    return kt.cuda(), exact


def _records(pages, slots):
    flat = pages.cpu().numpy().reshape(-1, 128, 68)
    return flat[slots // 128, slots % 128]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("rd,style", [(128, 0), (64, 0), (128, 1), (32, 1), (0, 0)])
@pytest.mark.parametrize("norm", [True, False])
def test_norm_rope_insert_matches_the_oracle(dtype, rd, style, norm):
    print(f"[gpu-test] norm_rope_insert {dtype} rd={rd} style={style} norm={norm}", flush=True)
    m = lib()
    rng = np.random.default_rng(rd + 7 * style + 3 * norm + (dtype == "bf16"))
    n, nb = 1000, 12
    k, exact = _rows(rng, n, dtype)
    slots = rng.permutation(nb * 128)[:n].astype(np.int64)
    pos = np.concatenate([rng.integers(0, 4096, size=n // 2),
                          rng.integers(0, 3_000_000, size=n - n // 2)]).astype(np.int64)
    w = rng.uniform(0.2, 2.0, size=128).astype(np.float32) if norm else None
    eps, base = 1e-6, 500000.0
    pages = torch.zeros(nb * 8704, dtype=torch.uint8, device="cuda")
    m.mi_idx_norm_rope_insert_mxfp4(
        k, torch.from_numpy(slots).cuda(), pages,
        norm_weight=None if w is None else torch.from_numpy(w).cuda(), norm_eps=eps,
        positions=torch.from_numpy(pos).cuda(), rotary_dim=rd, rope_base=base, rope_style=style)
    torch.cuda.synchronize()
    y = oracle.norm_rope_rows(exact, None if w is None else w.astype(np.float64), eps, pos, rd,
                              base, style)
    frac = checker.compare_encoded(_records(pages, slots), y)
    print(f"[gpu-test] exact records {frac:.4f}", flush=True)
    assert frac > 0.9


def test_plain_call_equals_the_insert():
    print("[gpu-test] norm_rope_insert without norm and rotation", flush=True)
    m = lib()
    rng = np.random.default_rng(3)
    k, exact = _rows(rng, 777, "fp32")
    slots = torch.from_numpy(rng.permutation(8 * 128)[:777].astype(np.int64)).cuda()
    a = torch.zeros(8 * 8704, dtype=torch.uint8, device="cuda")
    b = torch.zeros_like(a)
    m.mi_idx_insert_mxfp4(k, slots, a)
    m.mi_idx_norm_rope_insert_mxfp4(k, slots, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
