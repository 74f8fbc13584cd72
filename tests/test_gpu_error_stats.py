"""GPU parity of the error analysis (nvfp4_error_stats) against the oracle:
per-bin counts bit-exact; per-bin binary64 sums of identical per-element terms
within the reordering bound n * 2^-52 (both sides may sum in any order)."""
import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
nv = pytest.importorskip("nvfp4_block_quantization_amd")

pytestmark = pytest.mark.gpu


def say(msg: str) -> None:
    print(f"[gpu-errstats] {msg}", flush=True)


def to_gpu(x: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def check(got: np.ndarray, ref: np.ndarray, tag: str) -> None:
    assert np.array_equal(got[0], ref[0]), f"{tag}: counts {got[0]} vs {ref[0]}"
    tol = ref[0] * 2.0 ** -52 * np.abs(ref[1:]) + 1e-300
    bad = np.abs(got[1:] - ref[1:]) > tol
    assert not bad.any(), f"{tag}: sums differ in bins {np.argwhere(bad).tolist()[:5]}"


def run(x, block="1d", rht=False, mask=0, rule="none", cap=448.0, w=0.25, nb=26, tag=""):
    say(f"{tag}: {x.shape[0]}x{x.shape[1]} {x.dtype} block={block} rht={rht} rule={rule} w={w} nbins={nb}")
    xg = to_gpu(x)
    a = nv.amax(xg, rht=rht, rht_mask=mask)
    got = nv.error_stats(xg, a, block=block, rht=rht, rht_mask=mask, rule=rule, scale_cap=cap, bin_width=w, nbins=nb)
    torch.cuda.synchronize()
    A = oracle.amax(x, rht=rht, mask=mask)
    cfg = oracle.make_config(block=block, rht=rht, rht_mask=mask, rule=rule, cap=cap)
    ref = oracle.error_stats(x, cfg, A, w, nb)
    check(got.cpu().numpy(), ref, tag)
    return got.cpu().numpy(), ref


@pytest.mark.parametrize("rule", ["none", "mse", "mae", "maxerr"])
@pytest.mark.parametrize("path", ["1d", "2d", "1d-rht"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_error_stats_matrix(rule, path, dtype):
    x = workloads.generate(1 if dtype == "f32" else 5, 96, 208, seed=17)
    mask = 0x5A3C if path == "1d-rht" else 0
    run(x, block="2d" if path == "2d" else "1d", rht=path == "1d-rht", mask=mask, rule=rule,
        cap=448.0 if rule == "none" else 256.0, tag=f"matrix-{path}-{dtype}-{rule}")


def test_error_stats_bins_and_edges():
    x = workloads.generate(2, 64, 256, seed=1)
    run(x, w=0.5, nb=13, tag="w0.5")
    run(x, w=1.0, nb=1, tag="one-bin")
    run(x, w=0.125, nb=64, tag="64-bins")
    z = np.zeros((32, 64), np.float32)
    z[3, 5] = -2.5
    run(z, rule="mse", cap=256.0, tag="zeros")


@pytest.mark.parametrize("k", [2, 3, 4, 5])
def test_error_stats_full_size_workloads(k):
    """Each workload at full size on the GPU, against the oracle on a band of
    rows with the full tensor's amax (counts and sums of the band); the full
    tensor's counts sum to its size."""
    c = workloads.CONFIGS[k]
    mask = nv.rht_signs_from_seed(c["rht_seed"]) if c["rht"] else 0
    rule = "none"
    say(f"full workload {k}: generating {c['rows']}x{c['cols']}")
    x = workloads.inputs(c)
    xg = to_gpu(x)
    a = nv.amax(xg, rht=c["rht"], rht_mask=mask)
    got = nv.error_stats(xg, a, block=c["block"], rht=c["rht"], rht_mask=mask, rule=rule, scale_cap=448.0)
    torch.cuda.synchronize()
    g = got.cpu().numpy()
    assert g[0].sum() == c["rows"] * c["cols"]
    say(f"full workload {k}: oracle amax")
    A = oracle.amax(x, rht=c["rht"], mask=mask)
    assert np.float32(A).view(np.uint32) == a.cpu().numpy().view(np.uint32)[0]
    r0 = (c["rows"] // 2) // 16 * 16
    band = np.ascontiguousarray(x[r0:r0 + 64])
    say(f"full workload {k}: band rows {r0}:{r0 + 64}")
    bg = nv.error_stats(to_gpu(band), a, block=c["block"], rht=c["rht"], rht_mask=mask, rule=rule, scale_cap=448.0)
    ref = oracle.error_stats(band, oracle.make_config(block=c["block"], rht=c["rht"], rht_mask=mask, rule=rule,
                                                      cap=448.0), A)
    check(bg.cpu().numpy(), ref, f"workload{k}-band")
    del xg
    torch.cuda.empty_cache()
