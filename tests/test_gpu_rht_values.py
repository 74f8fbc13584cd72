"""The 16-point transform's binary32 values on the GPU against the oracle's,
bit for bit ("Pretraining Large Language Models with NVFP4", section 2b: the
gradient's blocks are multiplied by a randomized 16-point Hadamard matrix
before quantization).

The transformed values never leave the kernels, so they are read back through
the error analysis (nvfp4_error_stats), whose kernel transforms each block
with the same device routine as the quantize and amax kernels.  Each probe is
a 16x16 tensor whose only nonzero row is one block, built as the inverse
transform of 16 targets whose scaled magnitudes lie about 0.37 apart; with
bins 0.125 wide every transformed value then has a bin of its own (the zero
rows add exact zeros to bin 0), so each bin's binary64 sums hold exactly one
term: eps^2 with eps = fl(y - fl(v * d)), and the exact-scale reference's
eps*^2.  Rounding to the nearest grid point keeps y within half a step of
fl(v * d), so the subtraction is exact (Sterbenz) and eps^2 determines
|y - fl(v * d)| exactly: equal sums on both sides mean the same y, up to a
reflection about fl(v * d) that a rounding difference cannot produce.  The
probe's amax (max |y|, from the transform in the amax kernel) is compared too.
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
nv = pytest.importorskip("nvfp4_block_quantization_amd")

pytestmark = pytest.mark.gpu

W, NB = 0.125, 64


def say(msg: str) -> None:
    print(f"[gpu-rht] {msg}", flush=True)


def _hadamard16():
    H = np.array([[1.0]])
    for _ in range(4):
        H = np.block([[H, H], [H, -H]])
    return H


def probes(n: int, dtype: str, seed: int):
    """n probe tensors (16x16, one nonzero row) with their sign masks."""
    rng = np.random.default_rng(seed)
    H = _hadamard16()
    xs, masks = [], []
    for p in range(n):
        mask = int(rng.integers(0, 1 << 16))
        D = np.array([-1.0 if (mask >> i) & 1 else 1.0 for i in range(16)])
        mag = 0.3 + 0.37 * rng.permutation(16)
        t = mag * (1.0 + 0.01 * rng.uniform(-1, 1, 16)) * rng.choice([-1.0, 1.0], 16)
        t *= 2.0 ** int(rng.integers(-20, 20)) * rng.uniform(1.0, 2.0)
        x_row = D * (H @ t) / 4.0                      # the inverse transform of t: x = D H t / 4
        x = np.zeros((16, 16), np.float64)
        x[p % 16] = x_row
        x32 = x.astype(np.float32)
        if dtype == "bf16":
            b = x32.view(np.uint32)
            b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)  # nearest-even to bf16
            xs.append(b)
        else:
            xs.append(x32)
        masks.append(mask)
    return xs, masks


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_transform_values_are_bit_identical(dtype):
    n = 1024
    xs, masks = probes(n, dtype, seed=7 if dtype == "f32" else 8)
    say(f"{n} probe blocks, {dtype}: GPU amax + error statistics with the transform")
    host = np.stack(xs)
    xg = torch.from_numpy(host)
    if dtype == "bf16":
        xg = xg.view(torch.bfloat16)
    xg = xg.cuda()
    amax = torch.empty(n, dtype=torch.float32, device="cuda")
    stats = torch.empty((n, 3, NB), dtype=torch.float64, device="cuda")
    ws = torch.empty(nv.amax_workspace_bytes(16, 16), dtype=torch.uint8, device="cuda")
    for p in range(n):
        nv.amax(xg[p], rht=True, rht_mask=masks[p], out=amax[p:p + 1], workspace=ws)
        nv.error_stats(xg[p], amax[p:p + 1], rht=True, rht_mask=masks[p], rule="none", scale_cap=448.0,
                       bin_width=W, nbins=NB, out=stats[p])
    torch.cuda.synchronize()
    got_a = amax.cpu().numpy()
    got = stats.cpu().numpy()
    say("oracle side")
    checked = 0
    for p in range(n):
        A = oracle.amax(xs[p], rht=True, mask=masks[p])
        assert np.float32(A).view(np.uint32) == got_a[p].view(np.uint32), f"probe {p}: amax"
        cfg = oracle.make_config(rht=True, rht_mask=masks[p], rule="none", cap=448.0)
        ref = oracle.error_stats(xs[p], cfg, A, W, NB)
        assert np.array_equal(got[p][0], ref[0]), f"probe {p}: counts"
        nonzero_row = xs[p][p % 16].astype(np.float64)
        y = oracle.rht16(nonzero_row.astype(np.float32) if dtype == "f32" else
                         (xs[p][p % 16].astype(np.uint32) << 16).view(np.float32), masks[p])
        assert np.count_nonzero(y) == 16
        counts = ref[0].copy()
        counts[0] -= 240                             # the zero rows
        single = counts == 1
        # bins holding exactly one transformed value: its terms must agree to the bit
        for row in (1, 2):
            assert np.array_equal(got[p][row][single].view(np.uint64), ref[row][single].view(np.uint64)), \
                f"probe {p}: bin sums {row}"
        checked += int(single.sum())
    say(f"{checked} of {16 * n} transformed values compared exactly")
    assert checked >= 0.9 * 16 * n
