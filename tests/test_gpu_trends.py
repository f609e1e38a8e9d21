"""Monotone page scores through the GPU path: rising scores make every page a
new entry of every row's running top-15 (the selection's queues fill and
drain all along the walk, and every decode list is full); falling scores
make none after the first 15.  Exact scores, so ids must match the oracle
bit for bit."""

import numpy as np
import pytest

from tests import checker
from tests.gpu_common import run_gpu, run_oracle
from tests.trends import make_trend

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["trend_decode", "trend_prefill"])
@pytest.mark.parametrize("direction", [1, -1])
def test_monotone_scores(name, direction):
    print(f"[gpu-test] {name} direction {direction}", flush=True)
    w = make_trend(name, 0, direction)
    out, _, _, _, _ = run_gpu(w)
    ref, scores, L, _ = run_oracle(w)
    assert np.array_equal(out, ref)
    checker.compare(out, ref, scores, L)
    # the expected ids directly: the 15 newest pages, or pages 0..14
    for t in range(0, out.shape[0], 37):
        n = min(15, int(L[t]))
        want = (list(range(int(L[t]) - 1, int(L[t]) - 1 - n, -1)) if direction > 0
                else list(range(n)))
        assert out[t, 0, :n].tolist() == want
