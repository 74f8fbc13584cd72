"""nvfp4_amax_noalloc (the amax pass with the library's per-GPU scratch array
instead of a caller workspace) against nvfp4_amax, through the C ABI: the same
bits on two calls in a row, the second with a smaller input, for both input
dtypes, with and without the Hadamard transform, and on a non-default stream."""
import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
nv = pytest.importorskip("nvfp4_block_quantization_amd")

pytestmark = pytest.mark.gpu


def say(msg: str) -> None:
    print(f"[gpu-noalloc] {msg}", flush=True)


def to_gpu(x: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def bits(t: torch.Tensor) -> int:
    return int(np.float32(t.item()).view(np.uint32))


@pytest.mark.parametrize("kind,rht", [(5, False), (1, False), (4, True)])
def test_amax_noalloc_matches_amax_on_two_calls(kind, rht):
    mask = 0xB3E1 if rht else 0
    # a large input (the partial count at its 1024 cap), then a smaller one
    for rows, cols in ((8192, 4096), (48, 208)):
        say(f"kind {kind} rht {rht}: {rows}x{cols}")
        x = workloads.generate(kind, rows, cols, seed=21 + rows)
        xg = to_gpu(x)
        ref = nv.amax(xg, rht=rht, rht_mask=mask)
        got = nv.amax_noalloc(xg, rht=rht, rht_mask=mask)
        torch.cuda.synchronize()
        assert bits(got) == bits(ref), (rows, cols)
        assert bits(got) == int(np.float32(oracle.amax(x, rht=rht, mask=mask)).view(np.uint32))


def test_amax_noalloc_empty_and_other_stream():
    xg = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda")
    assert nv.amax_noalloc(xg).item() == 0.0
    s = torch.cuda.Stream()
    x = workloads.generate(2, 256, 512, seed=5)
    xg = to_gpu(x)
    with torch.cuda.stream(s):
        got = nv.amax_noalloc(xg, stream=s)
    s.synchronize()
    assert bits(got) == bits(nv.amax(xg))
