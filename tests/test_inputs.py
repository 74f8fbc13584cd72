"""The seeded input generator reproduces the recorded tensors bit for bit."""
import json
import os

import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "input_digests.json")


@pytest.mark.parametrize("k", ["1", "2", "3", "4", "5"])
def test_workload_input_digest(wl, k):
    rec = json.load(open(GOLDEN))[k]
    x = wl.inputs(wl.CONFIGS[int(k)], seed=0)
    assert list(x.shape) == rec["shape"] and str(x.dtype) == rec["dtype"]
    assert wl.digest(x) == rec["sha256"]
